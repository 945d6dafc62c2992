// Grouped SwiGLU expert GEMMs over the expert-sorted rows.
//
//   gate_up: g = rows . Wg^T, u = rows . Wu^T (+ per-expert bias),
//            h = silu(min(g, L)) * min(max(u, -L), L)          -> h (act dtype)
//   down:    y = h . Wd^T (+ per-expert bias)                   -> y (f32)
//
// [SF1073] = SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own DSpark draft
// (stacked on #1035)": commit notes on the DeepSeek-V4 family (clamped SwiGLU
// on routed and shared experts) and on the V4.1 converter (w1/w3 fused into
// gate_up_proj, w2 into down_proj; FP4 experts packed two codes per byte, low
// nibble first, one E8M0 scale per 32 inputs).  [MI143] = MoE-Infinity PR
// #143 "feat(dflash): converge DFlash spec-decode stack -> dev (supersedes
// #140)": output-major MXFP4 codes [E,N,K/2] / scales [E,N,K/32], used without
// a transpose; per-expert biases.  [SGL48763] = sglang PR #48763 "[Feat]
// dflash: Serve MoE FFN drafts for DFlash and DSpark": DraftMLP commit note
// (gate-up and down linears with silu or the clamped SwiGLU).
//
// bf16 / MXFP4 weights: weight-streaming MFMA kernels (tile.hpp).  A
// persistent grid walks the (active group, column tile) items; each item
// streams its weight rows once per pass of up to MT*16 rows.  The clamp value
// is read at run time, so any limit works (+inf = no clamp).
// f32 weights: plain FMA kernels, one thread per output column.
#include "kernels.hpp"
#include "tile.hpp"

namespace moe {

__device__ __forceinline__ float swiglu_clamped(float g, float u, float lim) {
  g = fminf(g, lim);
  u = fminf(fmaxf(u, -lim), lim);
  return g / (1.f + expf(-g)) * u;
}

struct GroupInfo {
  int g, nrows, row0;
};

__device__ __forceinline__ GroupInfo group_of(const ExpertGemmArgs &a, int gi) {
  GroupInfo r;
  if (a.counts) {
    r.g = a.active[gi];
    r.nrows = a.counts[r.g];
    r.row0 = a.offsets[r.g];
  } else {
    r.g = 0;
    r.nrows = a.single_rows;
    r.row0 = 0;
  }
  return r;
}

// ---------------------------------------------------------------------------
// Streaming grouped GEMM, bf16 or MXFP4 weights, bf16 activations.
//   GATE_UP: item = 16 gate rows j and the matching 16 up rows N + j of the
//            group's [2N, Kdim] matrix; epilogue SwiGLU (+clamp, + bias) -> h
//   down:    item = 32 rows of the group's [N, Kdim] matrix; epilogue
//            (+ bias) -> y f32
// With `direct_out` (one expert per token, no shared expert) the down
// epilogue writes the token's output row, weight applied, instead of y.
// ---------------------------------------------------------------------------
template <int MT, int WF, bool GATHER, bool GATE_UP, bool LO>
__global__ __launch_bounds__(kBlockThreads) void expert_stream(ExpertGemmArgs a) {
  __shared__ f32x4_t red[kSplitWaves * MT * 2 * 64];
  constexpr bool PFA = MT <= 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int n_groups = a.counts ? a.n_active[0] : 1;
  const int n_items = n_groups * a.n_tiles;
  const uint16_t *A = static_cast<const uint16_t *>(a.A);

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int gi = item / a.n_tiles, nt = item % a.n_tiles;
    const GroupInfo G = group_of(a, gi);

    int wr[2];  // this lane's two weight rows
    if constexpr (GATE_UP) {
      wr[0] = nt * 16 + lr;
      wr[1] = a.N + nt * 16 + lr;
    } else {
      wr[0] = nt * 32 + lr;
      wr[1] = nt * 32 + 16 + lr;
    }
    const uint16_t *wrow[2];
    const uint8_t *crow[2], *srow[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (WF == W_MXFP4) {
        crow[s] = static_cast<const uint8_t *>(a.W) + (size_t)G.g * a.w_stride + (size_t)wr[s] * (a.Kdim / 2);
        srow[s] = a.Wscale + (size_t)G.g * a.s_stride + (size_t)wr[s] * (a.Kdim / 32);
      } else {
        wrow[s] = static_cast<const uint16_t *>(a.W) + (size_t)G.g * a.w_stride + (size_t)wr[s] * a.Kdim;
      }
    }

    for (int m0 = 0; m0 < G.nrows; m0 += MT * 16) {
      const int mt_count = min(MT, (G.nrows - m0 + 15) / 16);
      const uint16_t *arow[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = min(m0 + mt * 16 + lr, G.nrows - 1);
        size_t ar;
        if constexpr (GATHER)
          ar = (size_t)(a.perm[G.row0 + r] / a.topk);
        else
          ar = (size_t)(G.row0 + r);
        arow[mt] = A + ar * a.Kdim;
      }
      const uint16_t *arow_lo[MT];
      if constexpr (LO) {  // down: rows of the low halves of h
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          arow_lo[mt] = static_cast<const uint16_t *>(a.A_lo) +
                        (size_t)(G.row0 + min(m0 + mt * 16 + lr, G.nrows - 1)) * a.Kdim;
      }
      f32x4_t acc[MT][2];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      if constexpr (WF == W_MXFP4)
        accum_mxfp4_pf<MT, 2, PFA, kSplitWaves, LO>(crow, srow, arow, mt_count, a.Kdim, wave, acc, 0, -1,
                                                   true, arow_lo);
      else
        accum_bf16_pf<MT, 2, PFA, kSplitWaves, LO>(wrow, arow, mt_count, a.Kdim, wave, acc, 0, -1, true,
                                                  arow_lo);
      splitk_merge<MT, 2>(acc, red, mt_count, wave);

      {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt < mt_count && (mt % kSplitWaves) == wave) {
            const int row = m0 + mt * 16 + lr;
            if (row < G.nrows) {
              if constexpr (GATE_UP) {
                const int col = nt * 16 + 4 * lg;
                float gb[4] = {0.f, 0.f, 0.f, 0.f}, ub[4] = {0.f, 0.f, 0.f, 0.f};
                if (a.bias) {
                  const uint16_t *b = static_cast<const uint16_t *>(a.bias) + (size_t)G.g * a.bias_stride;
#pragma unroll
                  for (int q = 0; q < 4; ++q) {
                    gb[q] = bf16_to_f32(b[col + q]);
                    ub[q] = bf16_to_f32(b[a.N + col + q]);
                  }
                }
                uint32_t hb[4], lb[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const float hv = swiglu_clamped(acc[mt][0][q] + gb[q], acc[mt][1][q] + ub[q], a.limit);
                  hb[q] = f32_to_bf16(hv);
                  lb[q] = f32_to_bf16(hv - bf16_to_f32(hb[q]));  // h = hi + lo to ~16 bits
                }
                const size_t off = (size_t)(G.row0 + row) * a.N + col;
                *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + off) =
                    make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                if (a.out_lo)
                  *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out_lo) + off) =
                      make_uint2(lb[0] | (lb[1] << 16), lb[2] | (lb[3] << 16));
              } else {
                int slot = 0;
                float wt = 0.f;
                if (a.direct_out) {  // one expert per token: out = weight * y
                  slot = a.perm[G.row0 + row];
                  wt = a.weights[slot];
                }
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                  const int col = nt * 32 + s * 16 + 4 * lg;
                  float4 v = make_float4(acc[mt][s][0], acc[mt][s][1], acc[mt][s][2], acc[mt][s][3]);
                  if (a.bias) {
                    const uint16_t *b = static_cast<const uint16_t *>(a.bias) + (size_t)G.g * a.bias_stride + col;
                    v.x += bf16_to_f32(b[0]);
                    v.y += bf16_to_f32(b[1]);
                    v.z += bf16_to_f32(b[2]);
                    v.w += bf16_to_f32(b[3]);
                  }
                  if (a.direct_out) {
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.direct_out) + (size_t)slot * a.N + col) =
                        make_uint2(f32_to_bf16(wt * v.x) | (f32_to_bf16(wt * v.y) << 16),
                                   f32_to_bf16(wt * v.z) | (f32_to_bf16(wt * v.w) << 16));
                  } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + (size_t)(G.row0 + row) * a.N + col) = v;
                  }
                }
              }
            }
          }
        }
      }
      __syncthreads();  // `red` and `last_unit` are reused by the next pass / unit
    }
  }
}

// ---------------------------------------------------------------------------
// f32 weights and activations: one thread per output column, rows looped.
// grid.y = group slot (>= the active count: idle).
// ---------------------------------------------------------------------------
template <bool GATHER>
__global__ __launch_bounds__(256) void gate_up_f32(ExpertGemmArgs a) {
  const int n_groups = a.counts ? a.n_active[0] : 1;
  if ((int)blockIdx.y >= n_groups) return;
  const GroupInfo G = group_of(a, blockIdx.y);
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  if (j >= a.N) return;
  const float *W = static_cast<const float *>(a.W) + (size_t)G.g * a.w_stride;
  const float *wg = W + (size_t)j * a.Kdim, *wu = W + (size_t)(a.N + j) * a.Kdim;
  const float *A = static_cast<const float *>(a.A);
  float gb = 0.f, ub = 0.f;
  if (a.bias) {
    const float *b = static_cast<const float *>(a.bias) + (size_t)G.g * a.bias_stride;
    gb = b[j];
    ub = b[a.N + j];
  }
  for (int r = threadIdx.x >> 6; r < G.nrows; r += 4) {
    const size_t ar = GATHER ? (size_t)(a.perm[G.row0 + r] / a.topk) : (size_t)(G.row0 + r);
    const float *x = A + ar * a.Kdim;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < a.Kdim; ++k) {
      g = fmaf(x[k], wg[k], g);
      u = fmaf(x[k], wu[k], u);
    }
    static_cast<float *>(a.out)[(size_t)(G.row0 + r) * a.N + j] = swiglu_clamped(g + gb, u + ub, a.limit);
  }
}

__global__ __launch_bounds__(256) void down_f32(ExpertGemmArgs a) {
  const int n_groups = a.counts ? a.n_active[0] : 1;
  if ((int)blockIdx.y >= n_groups) return;
  const GroupInfo G = group_of(a, blockIdx.y);
  const int n = blockIdx.x * 64 + (threadIdx.x & 63);
  if (n >= a.N) return;
  const float *w = static_cast<const float *>(a.W) + (size_t)G.g * a.w_stride + (size_t)n * a.Kdim;
  const float *A = static_cast<const float *>(a.A);
  const float bias = a.bias ? static_cast<const float *>(a.bias)[(size_t)G.g * a.bias_stride + n] : 0.f;
  for (int r = threadIdx.x >> 6; r < G.nrows; r += 4) {
    const float *h = A + (size_t)(G.row0 + r) * a.Kdim;
    float y = 0.f;
    for (int k = 0; k < a.Kdim; ++k) y = fmaf(h[k], w[k], y);
    static_cast<float *>(a.out)[(size_t)(G.row0 + r) * a.N + n] = y + bias;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

static int stream_grid(long items) {
  const long cap = 256L * 8;  // several resident workgroups per CU; the rest loop
  return (int)std::max(1L, std::min(items, cap));
}

static int pick_mt(int max_rows) {
  if (max_rows <= 16) return 1;
  if (max_rows <= 32) return 2;
  return 5;  // wider row tiles run out of registers; more rows take more passes
}

template <int MT, bool GATE_UP>
static void launch_stream_mt(ExpertGemmArgs a, WFormat wf, bool gather, int max_groups, int max_rows,
                             hipStream_t st) {
  const dim3 g(stream_grid((long)max_groups * a.n_tiles)), b(kBlockThreads);
  if constexpr (GATE_UP) {
    if (wf == W_MXFP4) {
      if (gather) hipLaunchKernelGGL((expert_stream<MT, W_MXFP4, true, true, false>), g, b, 0, st, a);
      else hipLaunchKernelGGL((expert_stream<MT, W_MXFP4, false, true, false>), g, b, 0, st, a);
    } else {
      if (gather) hipLaunchKernelGGL((expert_stream<MT, W_BF16, true, true, false>), g, b, 0, st, a);
      else hipLaunchKernelGGL((expert_stream<MT, W_BF16, false, true, false>), g, b, 0, st, a);
    }
  } else {  // the down projection reads h rows in expert order: no gather
    if (a.A_lo) {
      if (wf == W_MXFP4) hipLaunchKernelGGL((expert_stream<MT, W_MXFP4, false, false, true>), g, b, 0, st, a);
      else hipLaunchKernelGGL((expert_stream<MT, W_BF16, false, false, true>), g, b, 0, st, a);
    } else {
      if (wf == W_MXFP4) hipLaunchKernelGGL((expert_stream<MT, W_MXFP4, false, false, false>), g, b, 0, st, a);
      else hipLaunchKernelGGL((expert_stream<MT, W_BF16, false, false, false>), g, b, 0, st, a);
    }
  }
}

template <bool GATE_UP>
static void launch_stream(const ExpertGemmArgs &a, WFormat wf, int max_groups, int max_rows,
                          hipStream_t st) {
  const bool gather = GATE_UP && a.perm != nullptr;
  switch (pick_mt(max_rows)) {
    case 1: launch_stream_mt<1, GATE_UP>(a, wf, gather, max_groups, max_rows, st); break;
    case 2: launch_stream_mt<2, GATE_UP>(a, wf, gather, max_groups, max_rows, st); break;
    default: launch_stream_mt<5, GATE_UP>(a, wf, gather, max_groups, max_rows, st); break;
  }
}

hipError_t launch_gate_up(const ExpertGemmArgs &a, WFormat wf, int max_groups, int max_rows,
                          hipStream_t st) {
  if (max_groups <= 0 || max_rows <= 0) return hipSuccess;
  if (wf == W_F32) {
    const dim3 grid((a.N + 63) / 64, max_groups);
    if (a.perm) hipLaunchKernelGGL(gate_up_f32<true>, grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL(gate_up_f32<false>, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  launch_stream<true>(a, wf, max_groups, max_rows, st);
  return hipGetLastError();
}

hipError_t launch_down(const ExpertGemmArgs &a, WFormat wf, int max_groups, int max_rows,
                       hipStream_t st) {
  if (max_groups <= 0 || max_rows <= 0) return hipSuccess;
  if (wf == W_F32) {
    const dim3 grid((a.N + 63) / 64, max_groups);
    hipLaunchKernelGGL(down_f32, grid, dim3(256), 0, st, a);
    return hipGetLastError();
  }
  launch_stream<false>(a, wf, max_groups, max_rows, st);
  return hipGetLastError();
}

}  // namespace moe
