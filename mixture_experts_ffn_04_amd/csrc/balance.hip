// Load-balancing state of the router, on the device.
//
// [SF1073] = SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own DSpark draft
// (stacked on #1035)", commit notes:
//   - tokens_per_expert: an int64 count per expert to which every training
//     forward adds its kept slots (moe_token_mask);
//   - MoEBalancing, once per optimizer step: the pooled counts go to
//     update_expert_bias, the counts are reset, and moe/step_balance is
//     reported (1 for a uniform load, E / K when it has collapsed);
//   - update_expert_bias: one DeepSeek-V3 sign step with a zero-mean delta;
//     rate 0 keeps the bias fixed.
//
// balance_count: a histogram of the kept slots in LDS per workgroup, added to
// the int64 counts with one 64-bit vector atomic per non-empty bin (integer
// adds, so the result does not depend on their order).
// balance_update: one workgroup over all experts (E <= 1024): integer sums and
// the maximum, the signs sign(sum(c) - E * c_e) decided exactly on integers,
// the fp32 delta rate * (s_e - sum(s) / E) in that order, counts reset.
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kCountThreads = 256;
constexpr int kCountTokens = 1024;  // tokens per workgroup
constexpr int kUpdateThreads = 1024;

__global__ __launch_bounds__(kCountThreads) void balance_count(BalanceCountArgs a) {
  extern __shared__ int hist[];  // [E]
  for (int e = threadIdx.x; e < a.E; e += kCountThreads) hist[e] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kCountTokens;
  const int t1 = min(a.T, t0 + kCountTokens);
  const int n = (t1 - t0) * a.K;
  for (int i = threadIdx.x; i < n; i += kCountThreads) {
    const int t = t0 + i / a.K;
    if (a.mask && a.mask[t] == 0) continue;
    const int e = a.indices[(size_t)t0 * a.K + i];
    if ((unsigned)e < (unsigned)a.E) atomicAdd(&hist[e], 1);  // ids outside [0, E) are not counted
  }
  __syncthreads();
  for (int e = threadIdx.x; e < a.E; e += kCountThreads) {
    const int h = hist[e];
    if (h) atomicAdd(reinterpret_cast<unsigned long long *>(a.counts) + e, (unsigned long long)h);
  }
}

template <typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T *lds, Op op) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = op(v, __shfl_xor(v, off, 64));
  if (lane == 0) lds[wave] = v;
  __syncthreads();
  T r = lds[0];
  for (int w = 1; w < kUpdateThreads / 64; ++w) r = op(r, lds[w]);
  __syncthreads();  // lds is reused by the next reduction
  return r;
}

__global__ __launch_bounds__(kUpdateThreads) void balance_update(BalanceUpdateArgs a) {
#pragma clang fp contract(off)
  __shared__ long long red64[kUpdateThreads / 64];
  __shared__ int red32[kUpdateThreads / 64];
  const int e = threadIdx.x;
  const bool on = e < a.E;
  const long long c = on ? (long long)a.counts[e] : 0;
  const long long total = block_reduce(c, red64, [](long long x, long long y) { return x + y; });
  const long long cmax = block_reduce(c, red64, [](long long x, long long y) { return x > y ? x : y; });
  // s_e = sign(mean(c) - c_e) = sign(sum(c) - E * c_e), exact on integers
  const long long d = total - (long long)a.E * c;
  const int s = on ? (d > 0) - (d < 0) : 0;
  const int ssum = block_reduce(s, red32, [](int x, int y) { return x + y; });
  if (on) {
    if (a.bias && a.rate != 0.f) {
      const float m = (float)ssum / (float)a.E;
      const float delta = a.rate * ((float)s - m);
      a.bias[e] = a.bias[e] + delta;
    }
    a.counts[e] = 0;
  }
  if (e == 0 && a.balance)
    a.balance[0] = total == 0 ? 1.f : (float)((double)a.E * (double)cmax / (double)total);
}

}  // namespace

hipError_t launch_balance_count(const BalanceCountArgs &a, hipStream_t st) {
  if (a.T <= 0) return hipSuccess;
  const dim3 grid((a.T + kCountTokens - 1) / kCountTokens);
  hipLaunchKernelGGL(balance_count, grid, dim3(kCountThreads), (size_t)a.E * sizeof(int), st, a);
  return hipGetLastError();
}

hipError_t launch_balance_update(const BalanceUpdateArgs &a, hipStream_t st) {
  if (a.E <= 0 || a.E > kUpdateThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(balance_update, dim3(1), dim3(kUpdateThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
