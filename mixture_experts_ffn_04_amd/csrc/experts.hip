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
// This file holds the f32 path (f32 weights and activations): plain FMA
// kernels, one thread per output column, rows looped.  The bf16 and MXFP4
// paths are the streaming (stream.hip) and tiled (tiled.hip) MFMA kernels.
// The clamp value is read at run time, so any limit works (+inf = no clamp).
#include "kernels.hpp"

namespace moe {

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
    static_cast<float *>(a.out)[(size_t)(G.row0 + r) * a.N + j] = swiglu_exact(g + gb, u + ub, a.limit, a.act);
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

hipError_t launch_gate_up_f32(const ExpertGemmArgs &a, int max_groups, hipStream_t st) {
  if (max_groups <= 0) return hipSuccess;
  const dim3 grid((a.N + 63) / 64, max_groups);
  if (a.perm)
    enqueue_kernel(gate_up_f32<true>, grid, dim3(256), 0, st, a);
  else
    enqueue_kernel(gate_up_f32<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_down_f32(const ExpertGemmArgs &a, int max_groups, hipStream_t st) {
  if (max_groups <= 0) return hipSuccess;
  const dim3 grid((a.N + 63) / 64, max_groups);
  enqueue_kernel(down_f32, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
