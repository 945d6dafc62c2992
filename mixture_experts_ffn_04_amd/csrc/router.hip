// Router: fp32 logits, then score -> select -> routing_weights, one wavefront
// per token.
//
// [SF1033] = SpecForge PR #1033 "MoE FFN for DFlash-family drafts: the
// module", "Router" section (table rows score / select / routing_weights) and
// its commit note on the 1e-20 epsilon.  [SF1073] = SpecForge PR #1073 "MoE
// drafts: DeepSeek-V4.1's own DSpark draft (stacked on #1035)", commit notes on
// the selection-only fp32 expert_bias, on select receiving the shifted scores
// and on the DeepSeek-V4 family (sqrt-softplus scores).  [SGL48763] = sglang
// PR #48763 "[Feat] dflash: Serve MoE FFN drafts for DFlash and DSpark",
// commit note on the DraftMoE forward (fp32 logits into top-k).
#include "kernels.hpp"
#include "tile.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Logits, bf16 inputs.  Workgroup tile: 16 columns x MT*16 tokens over one
// slice of the hidden dimension (blockIdx.z).  Every MFMA step sums 32 exact
// bf16 products into a fresh f32 accumulator; the step results are added in
// fp64, so the only rounding left before the final one is the step's own
// (logits end within about one f32 ulp of the exactly rounded sum, which is
// what keeps the GPU's top-k on the oracle's side of near-ties).
// ---------------------------------------------------------------------------
// Logits, bf16 inputs, many tokens: a workgroup computes 64 tokens x 128
// columns over the whole hidden dimension, so each token row is read once
// per 128 columns (the narrow kernel above reads it once per 16).  Stages of
// 128 hidden elements of both operands go through LDS (XOR-swizzled 16-byte
// chunks); the next stage's loads are in registers while the current one is
// multiplied.  Wave w takes columns 32w .. 32w + 31 of the tile for all 64
// tokens.  Same arithmetic as the narrow kernel: every MFMA step (32 exact
// bf16 products in a fresh f32 accumulator) is added in fp64.
// ---------------------------------------------------------------------------
namespace {
constexpr int kLT = 64, kLC = 128, kLK = 128;  // tokens, columns, hidden elements per stage
__device__ __forceinline__ int lunit(int row, int ch) { return row * 16 + (ch ^ (row & 15)); }
}  // namespace

__global__ __launch_bounds__(256) void router_logits_tiled(LogitsArgs a) {
  __shared__ u32x4_t Xs[kLT * 16];   // 16 KB
  __shared__ u32x4_t Gs[kLC * 16];   // 32 KB
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int ncols = a.E + (a.sh_gate ? 1 : 0);
  const int c0 = blockIdx.x * kLC, m0 = blockIdx.y * kLT;
  const uint16_t *gate = static_cast<const uint16_t *>(a.gate);
  const uint16_t *x = static_cast<const uint16_t *>(a.x);

  // loads: unit j*256 + tid -> row (j*256 + tid) / 16, chunk tid % 16
  const int ch = tid & 15;
  const uint16_t *xs[kLT * 16 / 256], *gs[kLC * 16 / 256];
#pragma unroll
  for (int j = 0; j < kLT * 16 / 256; ++j)
    xs[j] = x + (size_t)min(m0 + j * 16 + (tid >> 4), a.T - 1) * a.H + ch * 8;
#pragma unroll
  for (int j = 0; j < kLC * 16 / 256; ++j) {
    const int c = c0 + j * 16 + (tid >> 4);
    const uint16_t *row;
    if (c < a.E) row = gate + (size_t)c * a.H;
    else if (c == a.E && a.sh_gate) row = static_cast<const uint16_t *>(a.sh_gate);
    else row = gate;  // padding column: any valid row, result discarded
    gs[j] = row + ch * 8;
  }
  u32x4_t xv[kLT * 16 / 256], gv[kLC * 16 / 256];
  auto gload = [&](int k0) {
#pragma unroll
    for (int j = 0; j < kLT * 16 / 256; ++j) xv[j] = load16(xs[j] + k0);
#pragma unroll
    for (int j = 0; j < kLC * 16 / 256; ++j) gv[j] = load16(gs[j] + k0);
  };
  auto lstore = [&]() {
#pragma unroll
    for (int j = 0; j < kLT * 16 / 256; ++j) Xs[lunit(j * 16 + (tid >> 4), ch)] = xv[j];
#pragma unroll
    for (int j = 0; j < kLC * 16 / 256; ++j) Gs[lunit(j * 16 + (tid >> 4), ch)] = gv[j];
  };

  double acc[2][4][4];  // [column fragment][token fragment][q]
#pragma unroll
  for (int cf = 0; cf < 2; ++cf)
#pragma unroll
    for (int tf = 0; tf < 4; ++tf)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[cf][tf][q] = 0.0;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

  const int nst = a.H / kLK;  // whole 128-element stages; the 32-element tail below
  if (nst > 0) gload(0);
  for (int s = 0; s < nst; ++s) {
    __syncthreads();  // the previous stage's operands are consumed
    lstore();
    __syncthreads();
    if (s + 1 < nst) gload((s + 1) * kLK);
#pragma unroll
    for (int q = 0; q < kLK / 32; ++q) {
      u32x4_t af[2], bf[4];
#pragma unroll
      for (int cf = 0; cf < 2; ++cf) af[cf] = Gs[lunit(wave * 32 + cf * 16 + lr, 4 * q + lg)];
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) bf[tf] = Xs[lunit(tf * 16 + lr, 4 * q + lg)];
#pragma unroll
      for (int cf = 0; cf < 2; ++cf)
#pragma unroll
        for (int tf = 0; tf < 4; ++tf) {
          const f32x4_t p = mfma_16x16x32(af[cf], bf[tf], zero);
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) acc[cf][tf][q2] += (double)p[q2];
        }
    }
  }
  // hidden-dimension tail (H % 128, a multiple of 32): one MFMA step per
  // 32 elements straight from global memory
  for (int k = nst * kLK; k < a.H; k += 32) {
    u32x4_t af[2], bf[4];
#pragma unroll
    for (int cf = 0; cf < 2; ++cf) {
      const int c = c0 + wave * 32 + cf * 16 + lr;
      const uint16_t *row = c < a.E ? gate + (size_t)c * a.H
                                    : (c == a.E && a.sh_gate ? static_cast<const uint16_t *>(a.sh_gate) : gate);
      af[cf] = load16(row + k + 8 * lg);
    }
#pragma unroll
    for (int tf = 0; tf < 4; ++tf) bf[tf] = load16(x + (size_t)min(m0 + tf * 16 + lr, a.T - 1) * a.H + k + 8 * lg);
#pragma unroll
    for (int cf = 0; cf < 2; ++cf)
#pragma unroll
      for (int tf = 0; tf < 4; ++tf) {
        const f32x4_t p = mfma_16x16x32(af[cf], bf[tf], zero);
#pragma unroll
        for (int q2 = 0; q2 < 4; ++q2) acc[cf][tf][q2] += (double)p[q2];
      }
  }
  // lane holds columns c0 + 32 wave + 16 cf + 4 lg + q2 of token m0 + 16 tf + lr
#pragma unroll
  for (int tf = 0; tf < 4; ++tf) {
    const int t = m0 + tf * 16 + lr;
    if (t >= a.T) continue;
#pragma unroll
    for (int cf = 0; cf < 2; ++cf)
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int c = c0 + wave * 32 + cf * 16 + 4 * lg + q2;
        if (c < ncols) a.partial[(size_t)t * a.ldl + c] = acc[cf][tf][q2];
      }
  }
}

// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(kBlockThreads) void router_logits_bf16(LogitsArgs a) {
  __shared__ double red[kSplitWaves * MT * 64 * 4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int ncols = a.E + (a.sh_gate ? 1 : 0);
  const int c0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * MT * 16;
  const int split = blockIdx.z;
  const uint16_t *gate = static_cast<const uint16_t *>(a.gate);
  const uint16_t *x = static_cast<const uint16_t *>(a.x);

  const int col = c0 + lr;
  const uint16_t *wrow;
  if (col < a.E)
    wrow = gate + (size_t)col * a.H;
  else if (col == a.E && a.sh_gate)
    wrow = static_cast<const uint16_t *>(a.sh_gate);
  else
    wrow = gate;  // padding column: any valid row, result discarded

  const int mt_count = min(MT, (a.T - m0 + 15) / 16);
  const uint16_t *arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = x + (size_t)min(m0 + mt * 16 + lr, a.T - 1) * a.H;

  double acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[mt][q] = 0.0;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};

  const int nblk = a.H / kKBlock;
  const int b0 = split * a.blocks_per_split;
  const int b1 = min(nblk, b0 + a.blocks_per_split);
  for (int b = b0 + wave; b < b1; b += kSplitWaves) {
    u32x4_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = load16(wrow + b * kKBlock + 32 * i + 8 * lg);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt < mt_count) {
        u32x4_t av[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) av[i] = load16(arow[mt] + b * kKBlock + 32 * i + 8 * lg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4_t p = mfma_16x16x32(w[i], av[i], zero);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[mt][q] += (double)p[q];
        }
      }
    }
  }
  if (split == a.n_split - 1) {  // 32-element tail of the hidden dimension
    const int ntail = (a.H % kKBlock) / 32;
    for (int t = wave; t < ntail; t += kSplitWaves) {
      const int k = nblk * kKBlock + 32 * t + 8 * lg;
      const u32x4_t w = load16(wrow + k);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt < mt_count) {
          const f32x4_t p = mfma_16x16x32(w, load16(arow[mt] + k), zero);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[mt][q] += (double)p[q];
        }
      }
    }
  }

  // merge the waves' partials in wave order
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    if (mt < mt_count)
#pragma unroll
      for (int q = 0; q < 4; ++q) red[((wave * MT + mt) * 64 + lane) * 4 + q] = acc[mt][q];
  __syncthreads();
  double *out = a.partial + (size_t)split * a.T * a.ldl;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < mt_count && (mt % kSplitWaves) == wave) {
      const int t = m0 + mt * 16 + lr;
      if (t < a.T) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          double v = red[((0 * MT + mt) * 64 + lane) * 4 + q];
#pragma unroll
          for (int w = 1; w < kSplitWaves; ++w) v += red[((w * MT + mt) * 64 + lane) * 4 + q];
          const int c = c0 + 4 * lg + q;
          if (c < ncols) out[(size_t)t * a.ldl + c] = v;
        }
      }
    }
  }
}

// Logits, f32 inputs: one thread per (token, column).  Products of two f32
// values are exact in fp64 and the fp64 sum of a few thousand of them is far
// inside one f32 ulp, so the rounded logit is the exactly rounded one.
__global__ __launch_bounds__(256) void router_logits_f32(LogitsArgs a) {
  const int ncols = a.E + (a.sh_gate ? 1 : 0);
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (long)a.T * ncols) return;
  const int t = (int)(id / ncols), c = (int)(id % ncols);
  const float *x = static_cast<const float *>(a.x) + (size_t)t * a.H;
  const float *w = c < a.E ? static_cast<const float *>(a.gate) + (size_t)c * a.H
                           : static_cast<const float *>(a.sh_gate);
  double acc = 0.0;
  for (int h = 0; h < a.H; ++h) acc = fma((double)x[h], (double)w[h], acc);
  a.partial[(size_t)t * a.ldl + c] = acc;
}

// ---------------------------------------------------------------------------
// Score, select, routing weights.  Lane l holds experts l + 64*j, j < J.
// ---------------------------------------------------------------------------

// (value, index) maximum over the wavefront: larger value wins, equal values
// go to the lower index.  `aux` rides along with the winner.
__device__ __forceinline__ void wave_argmax(float &v, int &idx, float &aux) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(v, off, kWave);
    const int oi = __shfl_xor(idx, off, kWave);
    const float oa = __shfl_xor(aux, off, kWave);
    if (ov > v || (ov == v && oi < idx)) {
      v = ov;
      idx = oi;
      aux = oa;
    }
  }
}

// Score, select and routing weights of token t, one wavefront: v[j] is the
// fp64 logit sum of expert lane + 64 j (valid ones), gate_logit the fp64
// logit of the shared-expert gate column.
template <int J>
__device__ __forceinline__ void select_token(const SelectArgs &a, int t, const double (&v)[J],
                                             double gate_logit) {
  const int lane = threadIdx.x & 63;
  const float NEG_INF = -__builtin_inff();

  // fp32 logits: the fp64 sum rounded once; the optional logit bias is one
  // f32 add after that ([SF941] "What")
  float l[J], s[J], c[J];
  bool valid[J];
#pragma unroll
  for (int j = 0; j < J; ++j) valid[j] = lane + 64 * j < a.E;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    if (valid[j]) {
      l[j] = (float)v[j];
      if (a.router_bias) l[j] += a.router_bias[e];
    } else {
      l[j] = NEG_INF;
    }
  }

  // scores ([SF1033] Router table, row score; [SF1073] DeepSeek-V4 family),
  // evaluated in fp64 from the f32 logits and rounded once to f32
  if (a.score_fn == 0) {  // softmax
    float m = NEG_INF;
#pragma unroll
    for (int j = 0; j < J; ++j) m = fmaxf(m, l[j]);
    m = wave_max(m);
    double z[J], part = 0.0;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      z[j] = valid[j] ? exp((double)l[j] - (double)m) : 0.0;
      part += z[j];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, kWave);
#pragma unroll
    for (int j = 0; j < J; ++j) s[j] = (float)(z[j] / part);
  } else if (a.score_fn == 1) {  // sigmoid
#pragma unroll
    for (int j = 0; j < J; ++j) s[j] = (float)(1.0 / (1.0 + exp(-(double)l[j])));
  } else {  // sqrt(softplus), overflow-free softplus
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const double v = (double)l[j];
      s[j] = (float)sqrt(fmax(v, 0.0) + log1p(exp(-fabs(v))));
    }
  }

  // unshifted scores out; selection values = scores + expert_bias ([SF1073])
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    if (valid[j]) {
      a.scores[(size_t)t * a.E + e] = s[j];
      c[j] = a.expert_bias ? s[j] + a.expert_bias[e] : s[j];
    } else {
      c[j] = NEG_INF;
    }
  }

  // group-limited selection ([SF1033] Router table, row select): keep the
  // topk_group groups with the largest top-2 sums, drop the other experts.
  if (a.n_group > 1) {
    const int gsize = a.E / a.n_group;
    uint64_t kept = 0;
    if (gsize == 32 && a.E == 64 * J) {
      // expert lane + 64 j is in group 2 j + lane / 32: each half-wavefront
      // holds one group per register, so one 5-step butterfly over the half
      // gives every group's top-2 at once; the other half's group scores come
      // with one exchange, and every lane ranks the 2J group scores itself
      // (larger sum first, lower group on equal sums)
      float b1[J], b2[J];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        b1[j] = c[j];
        b2[j] = NEG_INF;
      }
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) {
#pragma unroll
        for (int j = 0; j < J; ++j) {
          const float o1 = __shfl_xor(b1[j], off, kWave);
          const float o2 = __shfl_xor(b2[j], off, kWave);
          const float n1 = fmaxf(b1[j], o1);
          const float n2 = fmaxf(fminf(b1[j], o1), fmaxf(b2[j], o2));
          b1[j] = n1;
          b2[j] = n2;
        }
      }
      float gs[2 * J];
      const int hf = lane >> 5;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float mine = b1[j] + b2[j];
        const float other = __shfl_xor(mine, 32, kWave);
        gs[2 * j] = hf ? other : mine;
        gs[2 * j + 1] = hf ? mine : other;
      }
#pragma unroll
      for (int g = 0; g < 2 * J; ++g) {
        int rank = 0;
#pragma unroll
        for (int h = 0; h < 2 * J; ++h) rank += (gs[h] > gs[g] || (gs[h] == gs[g] && h < g)) ? 1 : 0;
        if (rank < a.topk_group) kept |= 1ull << g;
      }
    } else {
    float my_gscore = NEG_INF;  // lane g holds the score of group g
    for (int g = 0; g < a.n_group; ++g) {
      float b1 = NEG_INF, b2 = NEG_INF;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int e = lane + 64 * j;
        if (valid[j] && e / gsize == g) {
          const float v = c[j];
          if (v > b1) {
            b2 = b1;
            b1 = v;
          } else if (v > b2) {
            b2 = v;
          }
        }
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float o1 = __shfl_xor(b1, off, kWave);
        const float o2 = __shfl_xor(b2, off, kWave);
        const float n1 = fmaxf(b1, o1);
        const float n2 = fmaxf(fminf(b1, o1), fmaxf(b2, o2));
        b1 = n1;
        b2 = n2;
      }
      if (lane == g) my_gscore = b1 + b2;
    }
    for (int r = 0; r < a.topk_group; ++r) {
      float v = (lane < a.n_group && !((kept >> lane) & 1ull)) ? my_gscore : NEG_INF;
      int gi = lane < a.n_group ? lane : 1 << 30;
      float dummy = 0.f;
      wave_argmax(v, gi, dummy);
      kept |= 1ull << gi;
    }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      if (valid[j] && !((kept >> (e / gsize)) & 1ull)) c[j] = NEG_INF;
    }
  }

  // top-K in rounds of four picks (larger value first, lower id on equal
  // values): every lane keeps its best four untaken candidates, sorted; a
  // 6-step butterfly merges the lists (two sorted 4-lists -> the top four:
  // the better of A[q] and B[3 - q] is a bitonic sequence holding them,
  // sorted by two compare-exchange layers), and the four winners are the
  // next four picks.  Four times fewer dependent reductions than one
  // wavefront argmax per pick.
  // (K <= 2: one or two plain wavefront argmax rounds are shorter.)
  auto better = [](float va, int ia, float vb, int ib) { return va > vb || (va == vb && ia < ib); };
  uint32_t taken = 0;
  int my_idx = 0;
  if (a.K <= 2) {
    for (int k = 0; k < a.K; ++k) {
      // lane-local best; ids grow with j, so a strict '>' keeps the lower id
      float bv = NEG_INF, bs = 0.f;
      int bi = 1 << 30;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        if (valid[j] && !((taken >> j) & 1u) && (bi == (1 << 30) || c[j] > bv)) {
          bv = c[j];
          bi = lane + 64 * j;
        }
      }
      wave_argmax(bv, bi, bs);
      if (bi < a.E && (bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == k) my_idx = bi;
    }
  }
  for (int k0 = 0; a.K > 2 && k0 < a.K; k0 += 4) {
    float lv[4] = {NEG_INF, NEG_INF, NEG_INF, NEG_INF};
    int li[4] = {1 << 30, 1 << 30, 1 << 30, 1 << 30};
    auto cx = [&](int p, int q) {  // larger of positions p < q first
      if (better(lv[q], li[q], lv[p], li[p])) {
        const float tv = lv[p];
        const int ti = li[p];
        lv[p] = lv[q];
        li[p] = li[q];
        lv[q] = tv;
        li[q] = ti;
      }
    };
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (valid[j] && !((taken >> j) & 1u) && better(c[j], lane + 64 * j, lv[3], li[3])) {
        lv[3] = c[j];
        li[3] = lane + 64 * j;
        cx(2, 3);
        cx(1, 2);
        cx(0, 1);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      float ov[4];
      int oi[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ov[q] = __shfl_xor(lv[q], off, kWave);
        oi[q] = __shfl_xor(li[q], off, kWave);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (better(ov[3 - q], oi[3 - q], lv[q], li[q])) {
          lv[q] = ov[3 - q];
          li[q] = oi[3 - q];
        }
      }
      cx(0, 2);
      cx(1, 3);
      cx(0, 1);
      cx(2, 3);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (k0 + q < a.K) {
        if (li[q] < a.E && (li[q] & 63) == lane) taken |= 1u << (li[q] >> 6);
        if (lane == k0 + q) my_idx = li[q];
      }
    }
  }
  // the unshifted score of the lane's pick, from the lane that holds it
  float my_score = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const float sv = __shfl(s[j], my_idx & 63, kWave);
    if ((my_idx >> 6) == j) my_score = sv;
  }

  // routing weights from the unshifted scores ([SF1033] Router table, row
  // routing_weights): sum in k order, +1e-20, divide, then route_scale.
  float w = 0.f;
  if (a.norm) {
    float tot = 0.f;
    for (int k = 0; k < a.K; ++k) tot += __shfl(my_score, k, kWave);
    w = (my_score / (tot + 1e-20f)) * a.route_scale;
  } else {
    w = my_score * a.route_scale;
  }
  if (lane < a.K) {
    a.indices[(size_t)t * a.K + lane] = my_idx;
    a.weights[(size_t)t * a.K + lane] = w;
  }
  if (a.has_shared_gate && lane == 0) a.gamma[t] = (float)(1.0 / (1.0 + exp(-gate_logit)));
}

// Select from the logits kernel's fp64 partial sums (n_split slices of the
// hidden dimension, added in slice order).
template <int J>
__global__ __launch_bounds__(256) void router_select(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;  // whole wavefront leaves together
  const size_t slice = (size_t)a.T * a.ldl;
  const double *prow = a.partial + (size_t)t * a.ldl;
  double v[J];
#pragma unroll
  for (int j = 0; j < J; ++j) v[j] = lane + 64 * j < a.E ? prow[lane + 64 * j] : 0.0;
#pragma unroll 4
  for (int sp = 1; sp < a.n_split; ++sp) {
    double p[J];
#pragma unroll
    for (int j = 0; j < J; ++j) p[j] = lane + 64 * j < a.E ? prow[sp * slice + lane + 64 * j] : 0.0;
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] += p[j];
  }
  double g = 0.0;
  if (a.has_shared_gate) {
    g = prow[a.E];
    for (int sp = 1; sp < a.n_split; ++sp) g += prow[sp * slice + a.E];
  }
  select_token<J>(a, t, v, g);
}

// Logits and select in one kernel for few columns (E + gate <= 64) and few
// tokens: a workgroup of NT threads per token.  Lane groups of
// L = NT / next_pow2(columns) threads each own one column and split the hidden dimension in 8-element
// chunks, four chunks per step with independent accumulators (so several
// loads are in flight); every product of two bf16 (or f32) values is exact
// in fp64 and the sums are fp64.  Groups reduce through shuffles and LDS,
// then wave 0 scores and selects.  The fp32 logit is the fp64 sum rounded
// once.
template <bool BF16, int NT>
__global__ __launch_bounds__(NT) void router_fused(SelectArgs a) {
  constexpr int NW = NT / 64;
  __shared__ double colsum[NW][64];  // per wave, per column
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x;
  const int ncols = a.E + (a.has_shared_gate ? 1 : 0);
  int G = 1;
  while (G < ncols) G <<= 1;
  const int L = NT / G;  // threads per column
  const int col = tid / L, sub = tid % L;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  if (col < ncols) {
    const int step = L * 8;  // elements between a thread's chunks
    if constexpr (BF16) {
      const uint16_t *xr = static_cast<const uint16_t *>(a.x) + (size_t)t * a.H;
      const uint16_t *wr = col < a.E ? static_cast<const uint16_t *>(a.gate) + (size_t)col * a.H
                                     : static_cast<const uint16_t *>(a.sh_gate);
      int k = sub * 8;
      // U chunks per step: all loads issued before the first product
      auto steps = [&](auto unroll) {
        constexpr int U = decltype(unroll)::value;
        for (; k + (U - 1) * step < a.H; k += U * step) {
          u32x4_t xv[U], wv[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            xv[u] = load16(xr + k + u * step);
            wv[u] = load16(wr + k + u * step);
          }
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              acc[u & 3] = fma((double)bf16_lo(xv[u][q]), (double)bf16_lo(wv[u][q]), acc[u & 3]);
              acc[u & 3] = fma((double)bf16_hi(xv[u][q]), (double)bf16_hi(wv[u][q]), acc[u & 3]);
            }
        }
      };
      steps(std::integral_constant<int, 8>{});
      steps(std::integral_constant<int, 4>{});
      for (; k < a.H; k += step) {
        const u32x4_t xv = load16(xr + k), wv = load16(wr + k);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[0] = fma((double)bf16_lo(xv[q]), (double)bf16_lo(wv[q]), acc[0]);
          acc[0] = fma((double)bf16_hi(xv[q]), (double)bf16_hi(wv[q]), acc[0]);
        }
      }
    } else {
      const float *xr = static_cast<const float *>(a.x) + (size_t)t * a.H;
      const float *wr = col < a.E ? static_cast<const float *>(a.gate) + (size_t)col * a.H
                                  : static_cast<const float *>(a.sh_gate);
      for (int k = sub * 8; k < a.H; k += step) {
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q & 3] = fma((double)xr[k + q], (double)wr[k + q], acc[q & 3]);
      }
    }
  }
  double v = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  // reduce the column's threads: within a wave, then (columns wider than a
  // wave) across waves in LDS
  for (int off = 1; off < min(L, 64); off <<= 1) v += __shfl_xor(v, off, kWave);
  if (L >= 64) {
    if (lane == 0) colsum[wave][0] = v;
  } else if (sub == 0) {
    colsum[wave][(tid % 64) / L] = v;
  }
  __syncthreads();
  if (wave != 0) return;
  // column c's sum: waves own 64 / L columns each when L < 64, or one column
  // spread over L / 64 waves
  double cs = 0.0;
  if (lane < ncols) {
    if (L >= 64) {
      const int wpc = L / 64;  // waves per column
      for (int w = 0; w < wpc; ++w) cs += colsum[lane * wpc + w][0];
    } else {
      const int cpw = 64 / L;  // columns per wave
      cs = colsum[lane / cpw][lane % cpw];
    }
  }
  double vv[1];
  vv[0] = cs;
  const double g = a.has_shared_gate ? __shfl(cs, a.E, kWave) : 0.0;
  select_token<1>(a, t, vv, g);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

// The 64 x 128 tiled kernel from 256 tokens when there are at least 64
// columns; narrower problems keep the 16-column kernel with its split over
// the hidden dimension (it fills the chip where tiles would be few).
static bool router_logits_use_tiled(int T, int ncols) { return T >= 256 && ncols >= 64; }

// Row-tile width and number of hidden-dimension slices of the bf16 logits
// kernel for a problem (host side; the same numbers size the workspace).
void router_logits_plan(int T, int H, int ncols, bool bf16, int *mt, int *n_split,
                        int *blocks_per_split) {
  if (!bf16) {
    *mt = 1;
    *n_split = 1;
    *blocks_per_split = H / kKBlock + 1;
    return;
  }
  if (router_logits_use_tiled(T, ncols)) {  // one pass over the hidden dimension
    *mt = 0;
    *n_split = 1;
    *blocks_per_split = H / kKBlock + 1;
    return;
  }
  *mt = T <= 16 ? 1 : (T <= 256 ? 2 : 4);
  const int n_ct = (ncols + 15) / 16, n_rt = (T + *mt * 16 - 1) / (*mt * 16);
  const int nblk = H / kKBlock;
  const long base = std::max(1L, (long)n_ct * n_rt);
  int s = (int)std::max(1L, (512 + base - 1) / base);
  s = std::min(s, std::max(1, nblk / kSplitWaves));
  const int per = nblk > 0 ? (nblk + s - 1) / s : 0;
  *n_split = per > 0 ? (nblk + per - 1) / per : 1;
  *blocks_per_split = per;
}

hipError_t launch_router_logits(const LogitsArgs &a, bool bf16, hipStream_t st) {
  const int ncols = a.E + (a.sh_gate ? 1 : 0);
  if (a.T == 0) return hipSuccess;
  if (!bf16) {
    const long n = (long)a.T * ncols;
    hipLaunchKernelGGL(router_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  if (router_logits_use_tiled(a.T, ncols)) {
    if (a.n_split != 1) return hipErrorInvalidValue;
    const dim3 grid((ncols + kLC - 1) / kLC, (a.T + kLT - 1) / kLT);
    hipLaunchKernelGGL(router_logits_tiled, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  int mt, n_split, per;
  router_logits_plan(a.T, a.H, ncols, true, &mt, &n_split, &per);
  const dim3 block(kBlockThreads);
  const dim3 grid((ncols + 15) / 16, (a.T + mt * 16 - 1) / (mt * 16), n_split);
  if (mt == 1)
    hipLaunchKernelGGL(router_logits_bf16<1>, grid, block, 0, st, a);
  else if (mt == 2)
    hipLaunchKernelGGL(router_logits_bf16<2>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(router_logits_bf16<4>, grid, block, 0, st, a);
  return hipGetLastError();
}

// Fused when a token's padded row of products is short (next_pow2(columns)
// x H <= 32K elements): wider rows make each thread's load chain long enough
// that the split logits kernel plus select is faster.
bool router_fused_applies(int T, int H, int E, bool shared_gate) {
  const int ncols = E + (shared_gate ? 1 : 0);
  int G = 1;
  while (G < ncols) G <<= 1;
  return T <= 512 && ncols <= 64 && (long)G * H <= 32768;
}

hipError_t launch_router_select(const SelectArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + 3) / 4), block(256);
  if (a.x) {  // logits computed here, a workgroup per token
    if (!router_fused_applies(a.T, a.H, a.E, a.has_shared_gate)) return hipErrorInvalidValue;
    // wide rows (padded columns x hidden > 16K elements): 1024 threads, so a
    // thread's chain of dependent loads stays short
    int G = 1;
    while (G < a.E + (a.has_shared_gate ? 1 : 0)) G <<= 1;
    const bool wide = (long)G * a.H > 16384;
    if (a.x_bf16) {
      if (wide) hipLaunchKernelGGL((router_fused<true, 1024>), dim3(a.T), dim3(1024), 0, st, a);
      else hipLaunchKernelGGL((router_fused<true, 256>), dim3(a.T), block, 0, st, a);
    } else {
      if (wide) hipLaunchKernelGGL((router_fused<false, 1024>), dim3(a.T), dim3(1024), 0, st, a);
      else hipLaunchKernelGGL((router_fused<false, 256>), dim3(a.T), block, 0, st, a);
    }
    return hipGetLastError();
  }
  if (a.E <= 64)
    hipLaunchKernelGGL(router_select<1>, grid, block, 0, st, a);
  else if (a.E <= 128)
    hipLaunchKernelGGL(router_select<2>, grid, block, 0, st, a);
  else if (a.E <= 256)
    hipLaunchKernelGGL(router_select<4>, grid, block, 0, st, a);
  else if (a.E <= 512)
    hipLaunchKernelGGL(router_select<8>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(router_select<16>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
