// Host-side launchers of the gfx950 kernels (one per kernel family).  Each
// enqueues its kernels on `st` and returns the launch status.
#pragma once

#include "common.hpp"

namespace moe {

void router_logits_plan(int T, int H, int ncols, bool bf16, int *mt, int *n_split,
                        int *blocks_per_split);
hipError_t launch_router_logits(const LogitsArgs &a, bool bf16, hipStream_t st);
hipError_t launch_router_select(const SelectArgs &a, hipStream_t st);
// logits fused into the select kernel: up to 512 tokens, 64 columns and
// next_pow2(columns) x H <= 32K
bool router_fused_applies(int T, int H, int E, bool shared_gate);
hipError_t launch_permute(const PermuteArgs &a, hipStream_t st);

enum WFormat { W_F32 = 0, W_BF16 = 1, W_MXFP4 = 2 };

// f32 expert GEMMs (f32 weights and activations).  `max_groups` bounds the
// number of active groups (host-known); the kernels read the actual list.
hipError_t launch_gate_up_f32(const ExpertGemmArgs &a, int max_groups, hipStream_t st);
hipError_t launch_down_f32(const ExpertGemmArgs &a, int max_groups, hipStream_t st);

// LDS-staged weight-streaming grouped GEMM (small token counts).  Work items
// are (row chunk, column tile); max_chunks bounds the chunk count.
hipError_t launch_stream(const ExpertGemmArgs &a, bool gate_up, WFormat wf, long max_chunks, hipStream_t st);
// rows per chunk (16 or 32) for `slots` (token, expert) pairs over E experts
int stream_chunk_rows(long slots, int E);

// Tiled grouped GEMM (large token counts).  max_rows_total bounds the rows of
// all groups together, max_groups the number of groups.  queue: kTiledQueueInts
// tile counters of this launch, zero when it starts (left past the tile count).
constexpr int kTiledQueueInts = 8;
hipError_t launch_tiled(const TiledGemmArgs &t, bool gate_up, WFormat wf, long max_rows_total,
                        int max_groups, int32_t *queue, hipStream_t st);
int tiled_tile_rows();

// Large-tile grouped GEMM (experts with hundreds of rows: matrix-core bound).
// Activations, h and one expert's weights must each span less than 4 GiB.
// queue: kTiledQueueInts tile counters, zero when the launch starts.
hipError_t launch_bigtile(const TiledGemmArgs &t, bool gate_up, WFormat wf, long max_rows_total,
                          int max_groups, int32_t *queue, hipStream_t st);
int bigtile_rows();

// MXFP4 gate_up on the block-scaled matrix cores: the activations as two
// MXFP8 terms (q: [rows][K/32][hi 32 B | lo 32 B] E4M3, s: [rows][K/32] hi
// scale | lo scale << 8, E8M0), written by launch_mxfp8_split from bf16 rows.
struct MxActs {
  uint8_t *q;
  uint16_t *s;
};
hipError_t launch_mxfp8_split(const uint16_t *x, long rows, int K, const MxActs &xa, hipStream_t st);
// Whether the block-scaled large tile takes this product (reduction a
// multiple of 64 and at most 4096, scale array on 16 bytes).
bool bigtile_mx_scaled_applies(const TiledGemmArgs &t);
hipError_t launch_bigtile_mx_scaled(const TiledGemmArgs &t, const MxActs &xa, long max_rows_total, int max_groups,
                                    hipStream_t st);

hipError_t launch_combine(const CombineArgs &a, bool bf16_out, hipStream_t st);
hipError_t launch_fill_i32(int32_t *p, int32_t v, size_t n, hipStream_t st);

hipError_t launch_balance_count(const BalanceCountArgs &a, hipStream_t st);

// Workspace bytes of the backward; with `a` and `ws`, also points a's scratch
// arrays into ws.
size_t backward_layout(int T, int K, int E, int H, int I, int Is, BackwardArgs *a, char *ws);
hipError_t launch_backward(const BackwardArgs &a, hipStream_t st);
hipError_t launch_balance_update(const BalanceUpdateArgs &a, hipStream_t st);

}  // namespace moe
