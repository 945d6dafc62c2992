// Weighted combine: out[t] = sum_k weights[t,k] * y[row(t,k)] + gamma_t * ysh[t]
// in f32, k in order, then one rounding to the output format.
//
// [SF1033] = SpecForge PR #1033 "MoE FFN for DFlash-family drafts: the
// module": the routing_weights step yields the weights that combine the
// experts' outputs.  [SGL48763] = sglang PR #48763 "[Feat] dflash: Serve MoE
// FFN drafts for DFlash and DSpark": the optional sigmoid-gated shared expert
// is added to the routed sum (DraftMoE forward commit note).
#include "kernels.hpp"

namespace moe {

// grid: (column chunks of 1024, tokens); each thread owns 4 adjacent columns.
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void combine_rows(CombineArgs a) {
  const int t = blockIdx.y;
  const float gam = a.ysh ? (a.gamma ? a.gamma[t] : 1.f) : 0.f;
  {
    const int c = blockIdx.x * 1024 + threadIdx.x * 4;
    if (c >= a.H) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < a.K; ++k) {
      const float w = a.weights[(size_t)t * a.K + k];
      const int row = a.inv[(size_t)t * a.K + k];
      const float4 y = *reinterpret_cast<const float4 *>(a.y + (size_t)row * a.H + c);
      acc.x = fmaf(w, y.x, acc.x);
      acc.y = fmaf(w, y.y, acc.y);
      acc.z = fmaf(w, y.z, acc.z);
      acc.w = fmaf(w, y.w, acc.w);
    }
    if (a.ysh) {
      const float4 s = *reinterpret_cast<const float4 *>(a.ysh + (size_t)t * a.H + c);
      acc.x = fmaf(gam, s.x, acc.x);
      acc.y = fmaf(gam, s.y, acc.y);
      acc.z = fmaf(gam, s.z, acc.z);
      acc.w = fmaf(gam, s.w, acc.w);
    }
    if constexpr (BF16_OUT) {
      const uint2 p = make_uint2(f32_to_bf16(acc.x) | (f32_to_bf16(acc.y) << 16),
                                 f32_to_bf16(acc.z) | (f32_to_bf16(acc.w) << 16));
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(a.out) + (size_t)t * a.H + c) = p;
    } else {
      *reinterpret_cast<float4 *>(static_cast<float *>(a.out) + (size_t)t * a.H + c) = acc;
    }
  }
}

hipError_t launch_combine(const CombineArgs &a, bool bf16_out, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((a.H + 1023) / 1024, a.T);
  if (bf16_out)
    enqueue_kernel(combine_rows<true>, grid, dim3(256), 0, st, a);
  else
    enqueue_kernel(combine_rows<false>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
