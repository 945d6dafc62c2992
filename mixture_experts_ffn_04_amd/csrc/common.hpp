// Shared definitions of the gfx950 MoE FFN kernels: vector types, bf16
// conversion, the MFMA wrapper and the argument blocks the host launchers
// pass to the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 <-> f32
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Low / high bf16 of a packed pair, as f32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two f32 -> one packed bf16 pair (a in the low half), round to nearest
// even: the single gfx950 conversion instruction v_cvt_pk_bf16_f32; the
// same bits as f32_to_bf16 on every non-NaN input.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// The experts' SwiGLU on the clamped pre-activations g' = min(g, L),
// u' = clamp(u, -L, L):
//   act 0 (clamped SwiGLU): silu(g') * u'
//   act 1 (gpt-oss's swigluoai, as published with gpt-oss): g' sigmoid(1.702 g') (u' + 1)
// [SGL48763] DraftMLP commit note (silu, the clamped SwiGLU, swigluoai);
// [SF1073] DeepSeek-V4 family commit note (the clamp).
constexpr float kOaiAlpha = 1.702f;


// The SwiGLU clamps, min(g, L) and clip(u, -L, L), written as selects so that
// a NaN passes through as the framework's clamp passes it (the hardware's
// min and max return the other operand of a NaN).  L = +inf: no clamp.
__device__ __forceinline__ float clamp_hi(float v, float hi) { return v > hi ? hi : v; }
__device__ __forceinline__ float clamp_sym(float v, float lim) { return v > lim ? lim : (v < -lim ? -lim : v); }
// With the hardware's exp2 and reciprocal approximations (about 1 ulp each,
// so a few ulp of f32 on the result: far below the bf16 rounding that
// follows).  Large |g| behaves as the exact form: exp2 overflows to inf and
// the reciprocal to 0 (-> -0), or underflows to 0 (-> g).  For act 0 the
// scale factor is exactly -log2(e).
__device__ __forceinline__ float swiglu_fast(float g, float u, float lim, int act) {
  g = clamp_hi(g, lim);
  u = clamp_sym(u, lim);
  const float k = act ? kOaiAlpha * -1.4426950408889634f : -1.4426950408889634f;
  const float e = __builtin_amdgcn_exp2f(g * k);
  return g * __builtin_amdgcn_rcpf(1.f + e) * (act ? u + 1.f : u);
}

// The same with the library expf and an IEEE division.
__device__ __forceinline__ float swiglu_exact(float g, float u, float lim, int act) {
  g = clamp_hi(g, lim);
  u = clamp_sym(u, lim);
  return g / (1.f + expf(act ? -kOaiAlpha * g : -g)) * (act ? u + 1.f : u);
}

// ---------------------------------------------------------------------------
// MFMA: D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16), one wavefront.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each with the 8
// consecutive reduction elements 8*(l/16) .. 8*(l/16)+7; it receives
// D[4*(l/16) + q][l % 16], q = 0..3.  Any permutation of the reduction index
// applied to both operands gives the same product, which the kernels use to
// let each lane read longer contiguous runs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma_16x16x32(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16), one wavefront.  Lane l
// supplies row (l % 32) of A and column (l % 32) of B with the 8 consecutive
// reduction elements 8*(l/32) .. +7; it receives
// acc[i] = D[8*(i/4) + 4*(l/32) + i%4][l % 32], i = 0..15.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16_t mfma_32x32x16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Streaming (read-once) 16-byte load that does not displace reused lines.
__device__ __forceinline__ u32x4_t load_stream16(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
}
__device__ __forceinline__ u32x4_t load16(const void *p) {
  return *reinterpret_cast<const u32x4_t *>(p);
}

// ---------------------------------------------------------------------------
// Wave reductions (butterfly: every lane ends with the result; the order of
// the additions is fixed, so results are reproducible).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// ---------------------------------------------------------------------------
// Launch with optional timing events.  The measurement hook of the C ABI
// (moe_profile_stage) arms a start/stop pair just before a stage whose work is
// one kernel; that kernel's launch takes the pair, and the GPU records them
// at the kernel's own start and end (hipExtLaunchKernelGGL), with no extra
// packets between the kernel and its neighbours.  Thread-local, defined with
// the hook.
// ---------------------------------------------------------------------------
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents &pending_launch_events();

// Enqueues only; the caller reads the launch status (hipGetLastError).
template <typename K, typename... Args>
inline void enqueue_kernel(K kern, dim3 grid, dim3 block, size_t lds, hipStream_t st, Args... args) {
  LaunchEvents &ev = pending_launch_events();
  if (ev.start || ev.stop) {
    const LaunchEvents e = ev;
    ev = LaunchEvents{};
    hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, st, e.start, e.stop, 0u, args...);
  } else {
    hipLaunchKernelGGL(kern, grid, block, lds, st, args...);
  }
}

// ---------------------------------------------------------------------------
// Argument blocks
// ---------------------------------------------------------------------------

// Router logits: partial[s][t, c] = x[t, K_s] . gate[c, K_s] over the s-th
// slice K_s of the hidden dimension, for c < E, plus column E = x[t] .
// sh_gate when sh_gate is given.  fp64 partial sums, row stride ldl; the
// select kernel adds the n_split slices in order and rounds once to fp32.
struct LogitsArgs {
  const void *x;        // [T, H] act dtype
  const void *gate;     // [E, H]
  const void *sh_gate;  // [H] or null
  double *partial;      // [n_split][T][ldl]
  int T, H, E, ldl;
  int n_split;          // slices of the hidden dimension
  int blocks_per_split; // 128-element blocks per slice (the last takes the 32-element tail)
};

// Score / select / routing weights, one wavefront per token.
struct SelectArgs {
  const double *partial;     // [n_split][T][ldl] logit partial sums
  int n_split;
  // fused path (few columns and tokens): logits computed by the select
  // kernel itself from x, the gate and the shared-expert gate row; null x =
  // read the partial sums
  const void *x, *gate, *sh_gate;
  int H, x_bf16;
  const float *router_bias;  // [E] or null
  const float *expert_bias;  // [E] or null
  float *scores;             // [T, E]
  int32_t *indices;          // [T, K]
  float *weights;            // [T, K]
  float *gamma;              // [T] shared-expert gate (when has_shared_gate)
  int T, E, K, ldl;
  int score_fn, n_group, topk_group, norm;
  float route_scale;
  int has_shared_gate;
};

// Histogram / scan / scatter of the T*K slots by expert.
struct PermuteArgs {
  const int32_t *indices;  // [T*K]
  int32_t *counts;         // [E]
  int32_t *user_counts;    // [E] or null
  int32_t *offsets;        // [E+1]
  int32_t *active_all;     // [E] every expert with rows, ascending
  int32_t *n_active_all;   // [1]
  int32_t *mtile_prefix;   // [E+1] prefix over active_all of ceil(rows / tile_rows)
  int tile_rows;
  int32_t *mtile_prefix2;  // [E+1] the same for tile_rows2
  int tile_rows2;
  int4 *chunks;            // [n_slots + E] chunks of <= chunk_rows rows (ExpertGemmArgs::chunks)
  int32_t *n_chunks;       // [1]
  int chunk_rows;
  int32_t *perm;           // [T*K] row -> slot
  int32_t *inv;            // [T*K] slot -> row
  int n_slots, E;
};

// Grouped expert GEMM over row groups (one group per active expert, or one
// group of `single_rows` rows for the shared expert).
//   gate_up (SwiGLU epilogue): out h[row, j], j < N_half, from weight rows j
//           (gate) and N_half + j (up) of the group's [2*N_half, Kdim] matrix.
//   down (store epilogue):     out y[row, n] f32, n < N, from weight row n of
//           the group's [N, Kdim] matrix.
struct ExpertGemmArgs {
  // activation rows
  const void *A;            // direct: [rows, Kdim]; gather: x [T, Kdim]
  const int32_t *perm;      // gather mode: row -> slot (token = slot / topk)
  int topk;
  // row chunks (streaming kernels): {expert, first row, rows | (chunks of the
  // expert << 16), first chunk of the expert} per chunk of at most chunk_rows
  // rows; null = one group of single_rows rows cut into chunks of chunk_rows
  const int4 *chunks;
  const int32_t *n_chunks;  // [1]
  int chunk_rows;
  // groups
  const int32_t *counts;    // [E] rows per expert; null = single group
  const int32_t *offsets;   // [E+1]
  const int32_t *active;    // [E]
  const int32_t *n_active;  // [1]
  int single_rows;
  // weights
  const void *W;            // bf16/f32 values or MXFP4 codes
  const uint8_t *Wscale;    // MXFP4 scales
  size_t w_stride;          // per group, in elements (bf16/f32) or bytes (codes)
  size_t s_stride;          // per group, bytes of scales
  int Kdim;
  int N;                    // output columns (gate_up: N_half = I; down: H)
  int n_tiles;              // column tiles per group
  const void *bias;         // gate_up: [G, 2*N]; down: [G, N]; act dtype; or null
  size_t bias_stride;
  const void *A_lo;         // down with bf16 h: low halves of h (h = hi + lo); or null
  // output
  void *out;                // gate_up: h [rows, N] act dtype; down: y [rows, N] f32
  void *out_lo;             // gate_up with bf16 h: bf16(h - hi) [rows, N]; or null
  float limit;              // SwiGLU clamp (+inf = none)
  int act;                  // SwiGLU kind (moe_activation): 0 silu(g) u, 1 g sigmoid(1.702 g) (u + 1)
  // down only: write out[token] = weight * y (bf16) instead of y; valid when
  // every token has one expert and there is no shared expert
  void *direct_out;
  const float *weights;     // [T*K] routing weights by slot
  // streaming kernels, bf16 weights: a second segment of work items after the
  // grouped ones, one group of rows2 rows with operands of its own and no
  // bias or gather (the shared expert in the routed launch); rows2 = 0: none
  int rows2;
  const void *A2;           // [rows2, Kdim2] activation rows
  const void *A2_lo;        // down with bf16 h: low halves; or null
  const void *W2;           // gate_up [2*N2, Kdim2] or down [N2, Kdim2], bf16
  int Kdim2, N2, n_tiles2;
  void *out2, *out2_lo;     // as out / out_lo, [rows2, N2]
};

// Tiled grouped GEMM (large token counts): same operands and epilogues as
// ExpertGemmArgs; groups are walked through active_all / mtile_prefix.
struct TiledGemmArgs {
  ExpertGemmArgs g;
  const int32_t *active_all;
  const int32_t *n_active_all;
  const int32_t *mtile_prefix;
};

// out[t] = sum_k weights[t,k] * y[inv[t*K+k]] + gamma[t] * ysh[t]
struct CombineArgs {
  const float *y;        // [T*K, H]
  const int32_t *inv;    // [T*K]
  const float *weights;  // [T, K]
  const float *ysh;      // [T, H] or null
  const float *gamma;    // [T] or null (null = 1)
  void *out;             // [T, H] act dtype
  int T, H, K;
};

// counts[e] += #{(t, k) : indices[t,k] = e, mask[t] != 0}
struct BalanceCountArgs {
  const int32_t *indices;  // [T, K]
  const uint8_t *mask;     // [T] or null (every token kept)
  int64_t *counts;         // [E], accumulated
  int T, K, E;
};

// Backward of the layer (csrc/backward.hip).  Inputs, gradient outputs and
// the scratch arrays that backward_layout() carves from the workspace.
struct GradPtrs {
  float *dx, *dgate, *drouter_bias, *dw_gate_up, *dw_down, *db_gate_up, *db_down, *dsh_gate_up, *dsh_down,
      *dsh_gate;
};
struct BackwardArgs {
  int T, K, E, H, I, Is;
  int act_bf16, w_bf16, norm, score_fn;
  int act;  // SwiGLU kind (moe_activation)
  float limit, route_scale;
  const void *x, *dout, *gate_w, *w_gate_up, *w_down, *b_gate_up, *b_down, *sh_gate_up, *sh_down, *sh_gate;
  const float *scores;
  const int32_t *indices;
  GradPtrs g;
  // scratch
  int32_t *row_slot, *row_token, *row_expert, *slot_row, *counts, *offsets, *mtile_prefix;
  int32_t *blk;   // [slot blocks][E]: expert counts of each block, then its first row per expert
  int tile_rows;  // row height of the tiles that mtile_prefix counts
  float *part;    // partial products of split reductions
  float *colpart; // chunk sums of the column reductions
  float *slot_w, *row_w, *pre, *hact, *gd, *dpre, *dx_rows, *dweights, *dl, *dx_router;
  float *pre_s, *hact_s, *gd_s, *dpre_s, *dx_sh, *gamma, *dgam, *dz;
};

// step balance, bias sign step, counts reset
struct BalanceUpdateArgs {
  int64_t *counts;  // [E], zeroed
  float *bias;      // [E] or null
  float *balance;   // [1] or null
  float rate;
  int E;
};

}  // namespace moe
