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
// Logits, bf16 inputs: logits[t, c] = x[t] . gate[c] (c < E), column E =
// x[t] . sh_gate.  Workgroup tile: 16 columns x MT*16 tokens; products of
// bf16 are exact in f32, accumulation in f32 on the matrix cores.
// ---------------------------------------------------------------------------
template <int MT>
__global__ __launch_bounds__(kBlockThreads) void router_logits_bf16(LogitsArgs a) {
  __shared__ f32x4_t red[kSplitWaves * MT * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int ncols = a.E + (a.sh_gate ? 1 : 0);
  const int c0 = blockIdx.x * 16;
  const int m0 = blockIdx.y * MT * 16;
  const uint16_t *gate = static_cast<const uint16_t *>(a.gate);
  const uint16_t *x = static_cast<const uint16_t *>(a.x);

  const int col = c0 + lr;
  const uint16_t *wrow[1];
  if (col < a.E)
    wrow[0] = gate + (size_t)col * a.H;
  else if (col == a.E && a.sh_gate)
    wrow[0] = static_cast<const uint16_t *>(a.sh_gate);
  else
    wrow[0] = gate;  // padding column: any valid row, result discarded

  const int rows_left = a.T - m0;
  const int mt_count = min(MT, (rows_left + 15) / 16);
  const uint16_t *arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(m0 + mt * 16 + lr, a.T - 1);
    arow[mt] = x + (size_t)r * a.H;
  }
  f32x4_t acc[MT][1];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  accum_bf16<MT, 1>(wrow, arow, mt_count, a.H, wave, acc);
  splitk_merge<MT, 1>(acc, red, mt_count, wave);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    if (mt < mt_count && (mt % kSplitWaves) == wave) {
      const int t = m0 + mt * 16 + lr;
      if (t < a.T) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = c0 + 4 * lg + q;
          if (c < ncols) a.logits[(size_t)t * a.ldl + c] = acc[mt][0][q];
        }
      }
    }
  }
}

// Logits, f32 inputs: one thread per (token, column), f32 fused multiply-add
// in index order.
__global__ __launch_bounds__(256) void router_logits_f32(LogitsArgs a) {
  const int ncols = a.E + (a.sh_gate ? 1 : 0);
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (long)a.T * ncols) return;
  const int t = (int)(id / ncols), c = (int)(id % ncols);
  const float *x = static_cast<const float *>(a.x) + (size_t)t * a.H;
  const float *w = c < a.E ? static_cast<const float *>(a.gate) + (size_t)c * a.H
                           : static_cast<const float *>(a.sh_gate);
  float acc = 0.f;
  for (int h = 0; h < a.H; ++h) acc = fmaf(x[h], w[h], acc);
  a.logits[(size_t)t * a.ldl + c] = acc;
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

template <int J>
__global__ __launch_bounds__(256) void router_select(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;  // whole wavefront leaves together
  const float NEG_INF = -__builtin_inff();
  const float *lrow = a.logits + (size_t)t * a.ldl;

  float l[J], s[J], c[J];
  bool valid[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    valid[j] = e < a.E;
    l[j] = valid[j] ? lrow[e] : NEG_INF;
    if (valid[j] && a.router_bias) l[j] += a.router_bias[e];
  }

  // score ([SF1033] Router table, row score; [SF1073] DeepSeek-V4 family)
  if (a.score_fn == 0) {  // softmax
    float m = NEG_INF;
#pragma unroll
    for (int j = 0; j < J; ++j) m = fmaxf(m, l[j]);
    m = wave_max(m);
    float z[J], part = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      z[j] = valid[j] ? expf(l[j] - m) : 0.f;
      part += z[j];
    }
    const float tot = wave_sum(part);
#pragma unroll
    for (int j = 0; j < J; ++j) s[j] = z[j] / tot;
  } else if (a.score_fn == 1) {  // sigmoid
#pragma unroll
    for (int j = 0; j < J; ++j) s[j] = 1.f / (1.f + expf(-l[j]));
  } else {  // sqrt(softplus), overflow-free softplus
#pragma unroll
    for (int j = 0; j < J; ++j)
      s[j] = sqrtf(fmaxf(l[j], 0.f) + log1pf(expf(-fabsf(l[j]))));
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
    uint64_t kept = 0;
    for (int r = 0; r < a.topk_group; ++r) {
      float v = (lane < a.n_group && !((kept >> lane) & 1ull)) ? my_gscore : NEG_INF;
      int gi = lane < a.n_group ? lane : 1 << 30;
      float dummy = 0.f;
      wave_argmax(v, gi, dummy);
      kept |= 1ull << gi;
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int e = lane + 64 * j;
      if (valid[j] && !((kept >> (e / gsize)) & 1ull)) c[j] = NEG_INF;
    }
  }

  // top-K: K rounds of a wavefront argmax (largest value, lowest id on ties)
  uint32_t taken = 0;
  int my_idx = 0;
  float my_score = 0.f;
  for (int k = 0; k < a.K; ++k) {
    // lane-local best; ids grow with j, so a strict '>' keeps the lower id
    float bv = NEG_INF, bs = 0.f;
    int bi = 1 << 30;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (valid[j] && !((taken >> j) & 1u) && (bi == (1 << 30) || c[j] > bv)) {
        bv = c[j];
        bi = lane + 64 * j;
        bs = s[j];
      }
    }
    wave_argmax(bv, bi, bs);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == k) {
      my_idx = bi;
      my_score = bs;
    }
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
  if (a.has_shared_gate && lane == 0) a.gamma[t] = 1.f / (1.f + expf(-lrow[a.E]));
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

hipError_t launch_router_logits(const LogitsArgs &a, bool bf16, hipStream_t st) {
  const int ncols = a.E + (a.sh_gate ? 1 : 0);
  if (a.T == 0) return hipSuccess;
  if (!bf16) {
    const long n = (long)a.T * ncols;
    hipLaunchKernelGGL(router_logits_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  constexpr int MT = 4;
  dim3 grid((ncols + 15) / 16, (a.T + MT * 16 - 1) / (MT * 16));
  hipLaunchKernelGGL(router_logits_bf16<MT>, grid, dim3(kBlockThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_router_select(const SelectArgs &a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.T + 3) / 4), block(256);
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
