// Permutation of the T*K (token, k) slots by expert: per-expert counts (the
// kept-slot counts of SpecForge PR #1073 "MoE drafts: DeepSeek-V4.1's own
// DSpark draft (stacked on #1035)", tokens_per_expert commit note), exclusive
// offsets, the list of active experts with the prefixes of their row tiles
// for two tile heights (the tiled GEMMs), the table of row chunks (the
// streaming GEMM) and the row <->
// slot maps that the grouped expert GEMMs and the combine read.
//
// One workgroup: LDS histogram (integer atomics, so the counts are exact and
// order independent), one block scan of the five per-expert quantities,
// scatter through per-expert LDS cursors.  1024 threads in general; a single
// wavefront when there are at most 256 slots and 64 experts (the scan is then
// one wave's shuffles, and the launch and barriers of 16 waves are saved).  The order of the rows inside one
// expert depends on atomic timing; every row is computed independently of
// its position, and the combine reads rows through the slot -> row map, so
// the layer's results do not.
#include "../../include/moe_ffn.h"
#include "kernels.hpp"

namespace moe {

constexpr int kPermuteThreads = 1024;
constexpr int kPermuteHeld = 4;  // slots whose ids a thread keeps in registers
static_assert(MOE_MAX_EXPERTS <= kPermuteThreads, "one expert per thread in the scan");

// Inclusive scans of N ints per thread over the block (NT threads), all N in
// one pass (one set of barriers).
template <int N, int NT>
__device__ __forceinline__ void block_inclusive_scan(int (&v)[N], int (*wsum)[NT / 64]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int n = __shfl_up(v[i], off, kWave);
      if (lane >= off) v[i] += n;
    }
  }
  if constexpr (NT == 64) return;  // one wave: done
  if (lane == 63) {
#pragma unroll
    for (int i = 0; i < N; ++i) wsum[i][wave] = v[i];
  }
  __syncthreads();
  static_assert(NT == 64 || NT / 64 >= N, "a wave per scanned value");
  if (wave < N) {  // wave i scans the wave totals of value i
    int w = lane < NT / 64 ? wsum[wave][lane] : 0;
#pragma unroll
    for (int off = 1; off < NT / 64; off <<= 1) {
      const int n = __shfl_up(w, off, kWave);
      if (lane >= off) w += n;
    }
    if (lane < NT / 64) wsum[wave][lane] = w;
  }
  __syncthreads();
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] += wsum[i][wave - 1];
  }
}

template <int NT>
__global__ __launch_bounds__(NT) void permute_slots(PermuteArgs a) {
  __shared__ int hist[NT == 64 ? 64 : MOE_MAX_EXPERTS];
  __shared__ int wsum[5][NT / 64];
  const int tid = threadIdx.x;

  if (tid < a.E) hist[tid] = 0;
  // up to kHeld slots per thread keep their expert ids in registers for the
  // scatter below (no second read)
  constexpr int kHeld = kPermuteHeld;
  const bool held = a.n_slots <= kHeld * NT;
  int ids[kHeld];
#pragma unroll
  for (int j = 0; j < kHeld; ++j) {
    const int s = tid + j * NT;
    ids[j] = held && s < a.n_slots ? a.indices[s] : -1;
  }
  __syncthreads();
  if (held) {
#pragma unroll
    for (int j = 0; j < kHeld; ++j)
      if (ids[j] >= 0) atomicAdd(&hist[ids[j]], 1);
  } else {
    for (int s = tid; s < a.n_slots; s += NT) atomicAdd(&hist[a.indices[s]], 1);
  }
  __syncthreads();

  const int v = tid < a.E ? hist[tid] : 0;
  const int any = (tid < a.E && v > 0) ? 1 : 0;
  const int mtiles = (v + a.tile_rows - 1) / a.tile_rows;
  const int mtiles2 = (v + a.tile_rows2 - 1) / a.tile_rows2;
  const int nch = (v + a.chunk_rows - 1) / a.chunk_rows;
  int sc[5] = {v, any, mtiles, mtiles2, nch};
  block_inclusive_scan<5, NT>(sc, wsum);
  const int incl = sc[0], any_incl = sc[1], mt_incl = sc[2], mt2_incl = sc[3], ch_incl = sc[4];
  if (tid < a.E) {
    a.counts[tid] = v;
    if (a.user_counts) a.user_counts[tid] = v;
    a.offsets[tid] = incl - v;
    if (any) {
      a.active_all[any_incl - 1] = tid;
      a.mtile_prefix[any_incl] = mt_incl;
      a.mtile_prefix2[any_incl] = mt2_incl;
    }
    // {expert, first row, rows | chunks of the expert << 16, first chunk of the expert}
    for (int j = 0; j < nch; ++j)
      a.chunks[ch_incl - nch + j] = make_int4(tid, incl - v + j * a.chunk_rows,
                                              min(a.chunk_rows, v - j * a.chunk_rows) | (int)((unsigned)nch << 16), ch_incl - nch);
    hist[tid] = incl - v;  // becomes the scatter cursor
  }
  if (tid == NT - 1) {
    a.offsets[a.E] = incl;
    a.n_active_all[0] = any_incl;
    a.mtile_prefix[0] = 0;
    a.mtile_prefix2[0] = 0;
    a.n_chunks[0] = ch_incl;
  }
  __syncthreads();

  if (held) {
#pragma unroll
    for (int j = 0; j < kHeld; ++j) {
      if (ids[j] >= 0) {
        const int s = tid + j * NT;
        const int row = atomicAdd(&hist[ids[j]], 1);
        a.perm[row] = s;
        a.inv[s] = row;
      }
    }
  } else {
    for (int s = tid; s < a.n_slots; s += NT) {
      const int row = atomicAdd(&hist[a.indices[s]], 1);
      a.perm[row] = s;
      a.inv[s] = row;
    }
  }
}

__global__ void fill_i32(int32_t *p, int32_t v, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_permute(const PermuteArgs &a, hipStream_t st) {
  if (a.n_slots <= kPermuteHeld * 64 && a.E <= 64)
    enqueue_kernel(permute_slots<64>, dim3(1), dim3(64), 0, st, a);
  else
    enqueue_kernel(permute_slots<kPermuteThreads>, dim3(1), dim3(kPermuteThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int32_t v, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, v, n);
  return hipGetLastError();
}

}  // namespace moe
